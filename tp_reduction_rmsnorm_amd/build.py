"""Build step of the HIP library: compiles csrc/*.hip for gfx950 into
``libfused_reduce_norm.so`` next to this file.

    python tp_reduction_rmsnorm_amd/build.py

(run it as a file: importing it through the package would first load the
Python binding, which needs the library this builds).

Flags: -ffp-contract=off keeps every FP32 multiply and add separate (the
pages build their boundary file with FMA contraction disabled, vLLM PR
#62366 "Details"); hipcc's defaults keep FP32 divide and sqrt correctly
rounded and denormals IEEE.  Packed FP32 instructions are disabled.  Only
the frn_* entry points are exported.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfused_reduce_norm.so")
SOURCES = [os.path.join(CSRC, f) for f in ("frn_kernels.hip", "frn_shapes.hip", "frn_api.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Flags that decide the generated code (no paths, so a hash of them does not
# depend on where the repository is checked out).
CODEGEN_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden",
]
FLAGS = CODEGEN_FLAGS + [
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def build(out: str = LIB, extra=()) -> str:
    tmp = out + f".tmp{os.getpid()}"
    cmd = [HIPCC, *FLAGS, *extra, *SOURCES, "-o", tmp]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the GPU-only target feature; that warning is harmless
    noise = "'-packed-fp32-ops' is not a recognized feature for this target"
    msg = "\n".join(l for l in (proc.stdout + proc.stderr).splitlines() if noise not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{msg}")
    if msg.strip():
        print(msg, file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
