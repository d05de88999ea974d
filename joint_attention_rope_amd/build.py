"""Build the gfx950 HIP library libklein_attn.so in-tree with hipcc.

Usage: python -m joint_attention_rope_amd.build
"""

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libklein_attn.so")
SOURCES = ["api.cpp", "attn_fwd_bf16.hip", "attn_fwd_fp8.hip", "qkv_rope_proj.hip", "rope_apply.hip",
           "split_schedule.hip", "attn_bwd.hip", "noalloc.hip"]
# Device kernels never see NaN inputs on purpose (a NaN in q/k/v propagates to
# out either way), so min/max need no IEEE NaN canonicalisation.  The host
# argument checks (std::isfinite on descales) keep full NaN semantics.
KERNEL_FLAGS = {"attn_fwd_bf16.hip": ["-fno-honor-nans"], "attn_fwd_fp8.hip": ["-fno-honor-nans"],
                "attn_bwd.hip": ["-fno-honor-nans"]}
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # never let the compiler form packed fp32 VALU ops (v_pk_add/mul/fma_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines()
                    if "not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + err)
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose: bool = False) -> str:
    """Compile every source (always) and link libklein_attn.so."""
    tag = "%d" % os.getpid()
    objs = []
    try:
        for src in SOURCES:
            obj = os.path.join(CSRC, src + ".o" + tag)
            cflags = [f for f in FLAGS if f != "-shared"]
            _run([HIPCC, *cflags, *KERNEL_FLAGS.get(src, []), "-c", "-o", obj,
                  os.path.join(CSRC, src)], verbose)
            objs.append(obj)
        tmp = LIB + ".tmp" + tag
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
        os.replace(tmp, LIB)
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
