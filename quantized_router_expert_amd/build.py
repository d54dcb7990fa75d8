"""Build the gfx950 HIP library quantized_router_expert_amd/libmoe_decode.so.

hipcc compiles for gfx950 only.  Packed fp32 VALU instructions are disabled
(-packed-fp32-ops): hipcc would otherwise form v_pk_*_f32 from plain float
code, and this library keeps to scalar fp32/fp64 arithmetic.  No fast-math:
fp32 division and square root stay correctly rounded.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmoe_decode.so")
SOURCES = ["moe_kernels.hip", "moe_stack.hip", "moe_batch.hip", "moe_requant.hip", "moe_abi.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-fno-gpu-rdc", "-ffp-contract=off"]


def build(out=LIB, extra=None, verbose=False):
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    cmd = [HIPCC, *FLAGS, *(extra or []), *srcs, "-o", out + ".tmp"]
    r = subprocess.run(cmd, cwd=CSRC, capture_output=True, text=True)
    # the host pass does not know the gfx feature name; that warning is expected
    msgs = [l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
