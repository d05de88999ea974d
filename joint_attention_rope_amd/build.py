"""Build the gfx950 HIP library libklein_attn.so in-tree with hipcc.

Usage: python -m joint_attention_rope_amd.build
"""

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libklein_attn.so")
SOURCES = ["api.cpp", "attn_fwd_bf16.hip", "attn_fwd_fp8.hip", "rope_apply.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # never let the compiler form packed fp32 VALU ops (v_pk_add/mul/fma_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def build(verbose: bool = False) -> str:
    """Compile every source into libklein_attn.so (always rebuilds)."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, "-o", tmp, *[os.path.join(CSRC, s) for s in SOURCES]]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines()
                    if "not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + err)
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
